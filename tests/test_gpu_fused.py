"""GPU parity of the fused producers rms_norm_per_block_quant and
silu_and_mul_per_block_quant against the CPU oracle, through the C ABI.

RMSNorm: the kernel takes every precision decision the oracle takes (sum of
squares of bf16 values in fp64, 1/sqrt in fp64 rounded once to fp32, two
fp32 products, fp32 quotient by the scale).  The only freedom is the order
of the fp64 additions, so codes and scales must match bit for bit except in
a row whose fp64 1/rms (from the oracle) lies within the summation-order
bound of an fp32 rounding midpoint: such a row accepts either rounding.

SiLU-and-mul: the kernel's y is the float32 rounding of a float64 value
within 2^-51 of silu(g) u (exact g u times a correctly rounded float64
logistic table); the oracle rounds its own float64 value once.  Codes and
scales must match bit for bit, except in a group holding a value whose
oracle float64 lies within 2^-48 of a float32 rounding midpoint: such a
group accepts the oracle's group rule applied with either rounding of that
value.  The count of such values is printed and bounded.
"""
import numpy as np
import pytest

import fp8_blockwise_quantized_token_amd as fb
import oracle
from fp8_blockwise_quantized_token_amd import synth

from gpu_common import dev, host, say, to_dev, to_dev_bf16
from near_midpoint import assert_groups_match, assert_rms_rows_match

pytestmark = pytest.mark.gpu

EPS = np.float32(1e-10)


def _x(M, K, key, dist="normal_outlier"):
    return synth.activations_bf16(synth.Case("sweep", "fused", M, 128, K, dist, False, 500 + key))


def _gpu_rms(x, w, eps_norm, ue8m0):
    q, s = fb.rms_norm_quant(to_dev_bf16(x), to_dev(w), eps_norm=eps_norm, ue8m0=ue8m0)
    return host(q), host(s)


def _gpu_silu(x, ue8m0):
    q, s = fb.silu_and_mul_quant(to_dev_bf16(x), ue8m0=ue8m0)
    return host(q), host(s)


def _assert_exact(q, s, rq, rs, what):
    if not np.array_equal(s, rs):
        bad = np.argwhere(s != rs)[:5]
        raise AssertionError((what, "scales", [(tuple(i), s[tuple(i)], rs[tuple(i)]) for i in bad]))
    if not np.array_equal(q, rq):
        bad = np.argwhere(q != rq)[:5]
        raise AssertionError((what, "codes", [(tuple(i), q[tuple(i)], rq[tuple(i)]) for i in bad]))


def _assert_silu(q, s, x, what, eps=EPS, ue8m0=False, max_flag_rate=1e-5):
    """Exact parity with the oracle up to near-midpoint values (see above)."""
    y64 = oracle.silu_and_mul_values(x)
    n = assert_groups_match(q, s, y64, lambda y32: oracle.group_quant_f32(y32, eps=eps, ue8m0=ue8m0), what,
                            max_flag_rate=max_flag_rate)
    say("  near-midpoint values:", n, "of", y64.size)
    return n


def _assert_rms(q, s, x, w, eps_norm, what, eps=EPS, ue8m0=False):
    """Exact parity with the oracle up to rows whose 1/rms is next to a midpoint."""
    r64 = oracle.rms_norm_inv_rms(x, eps_norm=eps_norm)
    n = assert_rms_rows_match(q, s, r64, lambda rows, r32: oracle.rms_norm_apply(x[rows], w, r32, eps=eps,
                                                                                   ue8m0=ue8m0), what)
    if n:
        say("  rows with 1/rms next to a midpoint:", n, "of", x.shape[0])
    return n


# ----------------------------------------------------------------- RMSNorm

# (M, H) cover every kernel shape.  Up to 1024 rows (decode): four waves
# per row for H a multiple of 2048 (2048 .. 16384), two for 5120 and 7168,
# one otherwise (1536, 2560, 3584); beyond 1024 rows: one wave per row up to
# 4096, two up to 8192, four beyond.  Masked shapes for H not a multiple of
# 512 (128, 384, 640, 4224, 9216, 20480).  M covers 1, ragged multiples of
# the rows a workgroup holds, and enough rows that every resident workgroup
# walks several.
RMS_CASES = [(1, 128), (3, 384), (5, 640), (2, 1536), (7, 2048), (3, 2560), (2, 3584), (17, 4096),
             (4, 4224), (33, 5120), (2, 6144), (3, 7168), (9, 8192), (2, 9216), (3, 10240), (6, 12288),
             (2, 14336), (4, 16384), (2, 20480), (3, 32768), (301, 4096), (64, 2048), (1001, 5120),
             (4096, 1024), (2048, 4096), (1100, 8192), (1050, 6144), (1030, 16384), (1025, 7168)]


@pytest.mark.parametrize("M,H", RMS_CASES)
def test_rms_norm_quant_matches_oracle(M, H):
    x = _x(M, H, H % 97)
    w = synth.norm_weight_f32(H)
    for ue8m0 in (False, True):
        say("rms_norm_per_block_quant", M, H, "ue8m0" if ue8m0 else "fp32")
        q, s = _gpu_rms(x, w, 1e-6, ue8m0)
        _assert_rms(q, s, x, w, 1e-6, (M, H, ue8m0), ue8m0=ue8m0)


@pytest.mark.parametrize("M,H", [(8192, 4096), (4096, 5120), (16384, 2048)])
def test_rms_norm_quant_full_size(M, H):
    # Qwen3-8B / 32B / 1.7B hidden sizes at prefill token counts
    x = _x(M, H, 7)
    w = synth.norm_weight_f32(H)
    say("rms_norm_per_block_quant full size", M, H)
    q, s = _gpu_rms(x, w, 1e-6, False)
    _assert_rms(q, s, x, w, 1e-6, (M, H))


def test_rms_norm_quant_edge_rows():
    import torch
    H = 1024
    rows = np.zeros((6, H), np.float32)
    rows[1] = 3.0                                   # constant row
    rows[2, 100] = -96.0                            # one nonzero value
    rows[3] = 2.0 ** -60                            # tiny values: eps_norm dominates
    rows[4, ::2], rows[4, 1::2] = 448.0, -1e-3      # wide dynamic range
    rows[5] = np.where(np.arange(H) % 3 == 0, -0.0, 0.0)  # signed zeros
    x = synth.to_bf16_bits(rows)
    w = synth.norm_weight_f32(H)
    for eps_norm in (1e-6, 0.0, 1e-2):
        for ue8m0 in (False, True):
            if eps_norm == 0.0:
                xs, wn = x[1:5], w                  # the zero rows would divide by zero
            else:
                xs, wn = x, w
            say("rms edge rows", eps_norm, ue8m0)
            q, s = _gpu_rms(xs, wn, eps_norm, ue8m0)
            _assert_rms(q, s, xs, wn, eps_norm, ("edge", eps_norm, ue8m0), ue8m0=ue8m0)
    # M = 0 is a no-op
    q, s = fb.rms_norm_quant(torch.empty((0, H), dtype=torch.bfloat16, device=dev()), to_dev(w))
    assert q.shape == (0, H)


@pytest.mark.parametrize("M,H", [(5, 4096), (1200, 4096), (3, 640)])
def test_rms_norm_quant_smallest_eps(M, H):
    # eps at the accepted floor 2^-80: zero groups get the scale 2^-80 / 448,
    # and a group with amax just above eps (weights 2^-80) still matches the
    # oracle bit for bit (the shortcut divisions stay exact down there)
    x = _x(M, H, 13, dist="normal")
    x[0] = 0                                      # zero row: eps_norm only, zero groups
    x[1 % M, : H // 2] = 0                        # half a row of zero groups
    w = synth.norm_weight_f32(H)
    w[:128] = np.float32(2.0 ** -80)              # |x r| of a few units -> amax near 2^-79
    eps = np.float32(2.0 ** -80)
    for ue8m0 in (False, True):
        say("rms smallest eps", M, H, ue8m0)
        q, s = fb.rms_norm_quant(to_dev_bf16(x), to_dev(w), eps_norm=1e-6, eps=float(eps), ue8m0=ue8m0)
        _assert_rms(host(q), host(s), x, w, 1e-6, ("smallest eps", M, H, ue8m0), eps=eps, ue8m0=ue8m0)
        assert host(s)[0, 0] == (np.float32(2.0 ** -88) if ue8m0 else eps / np.float32(448))


def test_rms_norm_quant_strided_formats_and_padding():
    import torch
    M, H = 37, 1152
    G = H // 128
    x = _x(M, H, 11)
    w = synth.norm_weight_f32(H)
    big = np.zeros((M, H + 64), np.uint16)
    big[:, :H] = x
    xd = to_dev_bf16(big)[:, :H]
    wd = to_dev(w)
    for e8m0 in (False, True):
        for mn in (False, True):
            say("rms strided", "e8m0" if e8m0 else "fp32", "mn" if mn else "row")
            q = torch.full((M, H + 48), 0xAB, dtype=torch.uint8, device=dev())
            dt = torch.uint8 if e8m0 else torch.float32
            s = torch.full((G, M + 8) if mn else (M, G + 8), 0x5A if e8m0 else -1.0, dtype=dt, device=dev())
            sv = s[:, :M] if mn else s[:, :G]
            fb.fp8_rms_norm_per_block_quant(xd, wd, q[:, :H], sv, ue8m0=True, scale_e8m0=e8m0,
                                            scale_mn_major=mn)
            qh, sh = host(q), host(s)
            assert np.all(qh[:, H:] == 0xAB)
            got = sh[:, :M].T if mn else sh[:, :G]
            got_f = ((got.astype(np.uint32) << 23).view(np.float32)) if e8m0 else got
            _assert_rms(qh[:, :H], np.ascontiguousarray(got_f), x, w, 1e-6, ("strided", e8m0, mn), ue8m0=True)
            assert np.all((sh[:, M:] if mn else sh[:, G:]) == (0x5A if e8m0 else -1.0))


def _closest_quotient_weights(H, seed):
    """A weight row whose groups divide values that lie as close to an fp32
    rounding midpoint as fp32 operands allow.  With x = +-1 and eps_norm = 0
    the row's 1/rms is exactly 1 and y = +-w, so these are the quotients the
    producer divides: per group, one value A sets the scale s = RN(A / 448)
    (drawn until its significand S is odd), and the others are RN(M S 2^e)
    for odd 25-bit midpoint significands M with M S = +-r (mod 2^25), r odd
    and small, at quotient magnitudes 2^-6 .. 2^7."""
    g = np.random.Generator(np.random.PCG64(seed))
    w = np.empty(H, np.float32)
    scales = np.empty(H // 128, np.float32)
    for grp in range(H // 128):
        while True:
            a = np.float32(g.uniform(0.5, 4.0) * 2.0 ** int(g.integers(-8, 8)))
            sc = np.float32(a / np.float32(448))
            S = int(sc.view(np.uint32) & 0x7FFFFF) | 0x800000
            if S & 1:
                break
        inv = pow(S, -1, 1 << 25)
        vals = [a]
        r = 1
        while len(vals) < 128:
            for sg in (1, -1):
                M = (sg * r * inv) % (1 << 25)
                if M >= (1 << 24) and len(vals) < 128:
                    e = int(g.integers(-6, 7))
                    vals.append(np.float32(M * 2.0 ** (e - 24) * float(sc)))  # the 49-bit product rounded once
            r += 2
        v = np.array(vals, np.float32) * np.where(g.random(128) < 0.5, -1, 1).astype(np.float32)
        g.shuffle(v)
        w[grp * 128:(grp + 1) * 128] = v
        scales[grp] = sc
    return w, scales


@pytest.mark.parametrize("M,H", [(8, 4096), (1100, 4096), (8, 1536), (1100, 1536)])
def test_rms_norm_quant_division_at_the_closest_quotients(M, H):
    """The producers divide fp32 values by the group scale through a float64
    product; these quotients are the hardest for it (a reciprocal 2^-47 off
    already changes some of them), and every code must still be the one the
    oracle's IEEE division gives."""
    w, sc = _closest_quotient_weights(H, 700 + H)
    q_ref = (w / np.repeat(sc, 128)).astype(np.float32)
    d_off = (1.0 / np.repeat(sc, 128).astype(np.float64)) * (1 + 2.0 ** -47)
    assert np.any((w.astype(np.float64) * d_off).astype(np.float32) != q_ref), "cases are not hard"
    g = np.random.Generator(np.random.PCG64(M + H))
    x = np.where(g.random((M, H)) < 0.5, np.uint16(0xBF80), np.uint16(0x3F80)).astype(np.uint16)  # bf16 -1 / +1
    rq, rs = oracle.rms_norm_per_block_quant(x, w, eps_norm=0.0, eps=EPS)
    assert np.array_equal(rs, np.broadcast_to(sc, rs.shape)), "1/rms is not exactly 1"
    say("closest quotients", M, H)
    q, s = _gpu_rms(x, w, 0.0, False)
    _assert_exact(q, s, rq, rs, ("closest quotients", M, H))


# ------------------------------------------------------------ SiLU and mul

SILU_CASES = [(1, 128), (3, 256), (5, 384), (64, 6144), (7, 12288), (2, 25600), (129, 1024)]


@pytest.mark.parametrize("M,I", SILU_CASES)
def test_silu_and_mul_quant_matches_oracle(M, I):
    x = _x(M, 2 * I, I % 89)
    for ue8m0 in (False, True):
        say("silu_and_mul_per_block_quant", M, I, "ue8m0" if ue8m0 else "fp32")
        q, s = _gpu_silu(x, ue8m0)
        _assert_silu(q, s, x, (M, I, ue8m0), ue8m0=ue8m0)


@pytest.mark.parametrize("M,I", [(8192, 12288), (4096, 25600)])
def test_silu_and_mul_quant_full_size(M, I):
    # Qwen3-8B / 32B intermediate sizes at prefill token counts
    x = _x(M, 2 * I, 3)
    say("silu_and_mul_per_block_quant full size", M, I)
    for ue8m0 in (False, True):
        q, s = _gpu_silu(x, ue8m0)
        _assert_silu(q, s, x, (M, I, ue8m0), ue8m0=ue8m0)


def test_silu_and_mul_quant_special_gates():
    # large positive gates (silu = gate), very negative gates (signed zeros),
    # zero gates, mixed in one row: exact agreement expected
    I = 512
    gen = synth.generator(51)
    gate = np.empty((4, I), np.float32)
    gate[0] = gen.uniform(40.0, 200.0, I)
    gate[1] = -gen.uniform(100.0, 3e4, I)
    gate[2] = 0.0
    gate[3, ::2], gate[3, 1::2] = 64.0, -90.0
    up = gen.standard_normal((4, I)).astype(np.float32)
    x = synth.to_bf16_bits(np.concatenate([gate, up], axis=1))
    for ue8m0 in (False, True):
        say("silu special gates", ue8m0)
        q, s = _gpu_silu(x, ue8m0)
        rq, rs = oracle.silu_and_mul_per_block_quant(x, ue8m0=ue8m0)
        _assert_exact(q, s, rq, rs, ("special", ue8m0))
        assert _assert_silu(q, s, x, ("special", ue8m0), ue8m0=ue8m0) == 0


@pytest.mark.parametrize("M,I", [(4, 1024), (600, 12288)])
def test_silu_and_mul_quant_smallest_eps(M, I):
    # eps at the floor 2^-80: zero gates give zero groups with the scale
    # 2^-80 / 448 exactly, and a row with gate 2^-40 and up near 2^-40 has
    # group amaxes just above eps
    x = _x(M, 2 * I, 17, dist="normal")
    x[0, :I] = 0
    gen = synth.generator(52)
    x[1 % M, :I] = synth.to_bf16_bits(np.full((1, I), 2.0 ** -40, np.float32))[0]
    x[1 % M, I:] = synth.to_bf16_bits((gen.standard_normal((1, I)) * 2.0 ** -40).astype(np.float32))[0]
    eps = np.float32(2.0 ** -80)
    for ue8m0 in (False, True):
        say("silu smallest eps", M, I, ue8m0)
        q, s = fb.silu_and_mul_quant(to_dev_bf16(x), eps=float(eps), ue8m0=ue8m0)
        rq, rs = oracle.silu_and_mul_per_block_quant(x, eps=eps, ue8m0=ue8m0)
        q, s = host(q), host(s)
        assert np.all(s[0] == rs[0]) and np.all(q[0] == rq[0])  # zero groups: exact
        _assert_silu(q, s, x, ("silu smallest eps", M, I, ue8m0), eps=eps, ue8m0=ue8m0)
        assert np.all(rs[1 % M] < np.float32(2.0 ** -75))


def test_silu_and_mul_quant_strided_formats_and_padding():
    import torch
    M, I = 21, 640
    G = I // 128
    x = _x(M, 2 * I, 13)
    big = np.zeros((M, 2 * I + 32), np.uint16)
    big[:, :2 * I] = x
    xd = to_dev_bf16(big)[:, :2 * I]
    rq, rs = oracle.silu_and_mul_per_block_quant(x, ue8m0=True)
    for e8m0 in (False, True):
        for mn in (False, True):
            say("silu strided", "e8m0" if e8m0 else "fp32", "mn" if mn else "row")
            q = torch.full((M, I + 16), 0xAB, dtype=torch.uint8, device=dev())
            dt = torch.uint8 if e8m0 else torch.float32
            s = torch.full((G, M + 8) if mn else (M, G + 8), 0x5A if e8m0 else -1.0, dtype=dt, device=dev())
            sv = s[:, :M] if mn else s[:, :G]
            fb.fp8_silu_and_mul_per_block_quant(xd, q[:, :I], sv, ue8m0=True, scale_e8m0=e8m0,
                                                scale_mn_major=mn)
            qh, sh = host(q), host(s)
            assert np.all(qh[:, I:] == 0xAB)
            got = sh[:, :M].T if mn else sh[:, :G]
            got_f = ((got.astype(np.uint32) << 23).view(np.float32)) if e8m0 else got
            _assert_silu(qh[:, :I], np.ascontiguousarray(got_f), x, ("strided", e8m0, mn), ue8m0=True)
            assert np.all((sh[:, M:] if mn else sh[:, G:]) == (0x5A if e8m0 else -1.0))


def test_silu_and_mul_quant_table_path_all_gate_ranges():
    # large enough for the sigmoid-table path; gates cover every table
    # region: below 2^-25, each binade up to 128, beyond 128, zeros, both signs
    M, I = 2048, 8192
    gen = synth.generator(52)
    mag = np.exp2(gen.uniform(-40.0, 10.0, (M, I))).astype(np.float32)
    gate = np.where(gen.random((M, I)) < 0.5, -mag, mag).astype(np.float32)
    gate[:, ::97] = 0.0
    up = gen.standard_normal((M, I)).astype(np.float32)
    x = synth.to_bf16_bits(np.concatenate([gate, up], axis=1))
    # Gates of 2^-24 .. 2^-16 make exact ties common: there silu(g) u is
    # g u / 2 + g^2 u / 4 up to a relative g^2 / 12, and both terms have few
    # significant bits, so the value often lies within about 2^-70 of a float32
    # midpoint, closer than either float64 evaluation can resolve.  Those
    # values are flagged (about 2.4e-4 of this input) and accept either rounding.
    for ue8m0 in (False, True):
        say("silu table path, all gate ranges", M, I, ue8m0)
        q, s = _gpu_silu(x, ue8m0)
        _assert_silu(q, s, x, ("table path", ue8m0), ue8m0=ue8m0, max_flag_rate=1e-3)


def test_silu_and_mul_quant_row_chunks_with_a_wide_pitch():
    # a row pitch of 2^27 elements limits one launch to 15 rows (32-bit
    # offsets), so 40 rows take three launches; only the first 2I columns of
    # each row are read
    import torch
    M, I = 40, 256
    pitch = 1 << 27
    x = _x(M, 2 * I, 17)
    big = torch.empty((M, pitch), dtype=torch.bfloat16, device=dev())
    big[:, :2 * I] = to_dev_bf16(x)
    xd = big[:, :2 * I]
    assert xd.stride(0) == pitch
    for ue8m0 in (False, True):
        say("silu wide pitch, chunked rows", M, I, pitch, ue8m0)
        q, s = fb.silu_and_mul_quant(xd, ue8m0=ue8m0)
        q, s = host(q), host(s)
        _assert_silu(q, s, x, ("wide pitch", ue8m0), ue8m0=ue8m0)
    del big
    torch.cuda.empty_cache()


# ------------------------------------------- producers feeding the GEMM


@pytest.mark.parametrize("M", [1, 24, 300])
def test_producers_feed_the_block_gemm(M):
    """The MLP of a Qwen3-8B layer on the hot path: RMSNorm + group quant ->
    gate_up GEMM -> SiLU-and-mul + group quant -> down GEMM, every step in
    the library, against the oracle's chain of the same steps (each GEMM
    output rounded to bf16 as the library's is).  The codes feeding each
    GEMM are compared first (RMSNorm: bit-exact; SiLU-and-mul: to its
    tolerance), then the final output to the GEMM tolerance, on the oracle's
    own inputs to each GEMM so that no difference carries over."""
    import torch
    from gpu_common import assert_close, oracle_weight, sample_rows
    H, I = 4096, 12288
    x = _x(M, H, 23)
    w_norm = synth.norm_weight_f32(H)
    # gate_up weight [2I, H], down weight [H, I], quantized by the oracle
    qgu, sgu = oracle_weight(2 * I, H, False)
    qdn, sdn = oracle_weight(H, I, False)
    say("mlp chain", M)
    # library chain
    qa, sa = fb.rms_norm_quant(to_dev_bf16(x), to_dev(w_norm))
    h = fb.block_gemm(qa, sa, to_dev(qgu), to_dev(sgu))
    qh, shh = fb.silu_and_mul_quant(h)
    y = fb.block_gemm(qh, shh, to_dev(qdn), to_dev(sdn))
    # oracle chain
    rqa, rsa = oracle.rms_norm_per_block_quant(x, w_norm)
    _assert_rms(host(qa), host(sa), x, w_norm, 1e-6, ("mlp rmsnorm", M))
    rows = sample_rows(M, 8, key=M)
    h_ref = oracle.block_gemm(rqa, rsa, qgu, sgu, rows=rows)
    assert_close(host(h)[rows].astype(np.float64), h_ref, "gate_up")
    # the library's own bf16 h (within tolerance of the oracle) feeds both sides
    hb = h.view(torch.int16).cpu().numpy().view(np.uint16)
    rqh, rsh = oracle.silu_and_mul_per_block_quant(hb)
    _assert_silu(host(qh), host(shh), hb, ("mlp silu", M))
    y_ref = oracle.block_gemm(host(qh), host(shh), qdn, sdn, rows=rows)
    assert_close(host(y)[rows].astype(np.float64), y_ref, "down")
