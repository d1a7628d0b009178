"""GPU parity of the quantizers and the encoder against the CPU oracle.

Quantized bytes and scales must match the oracle bit for bit.  Inputs are the
seeded synthetic activations/weights of every workload (synth.py), the
hand-worked groups of tests/golden, every bf16 value, and every fp32 pattern
in [0, 448] for the bare encoder.
"""
import os

import numpy as np
import pytest

import fp8_blockwise_quantized_token_amd as fb
import oracle
from fp8_blockwise_quantized_token_amd import synth

from gpu_common import dev, host, oracle_weight, say, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

EPS = np.float32(1e-10)


def _gpu_encode(f: np.ndarray) -> np.ndarray:
    import torch
    t = to_dev(f)
    q = torch.empty(t.shape, dtype=torch.uint8, device=dev())
    fb.fp8_e4m3_encode(t, q)
    return q.cpu().numpy()


def test_encode_every_nonnegative_fp32_up_to_448():
    top = int(np.float32(448.0).view(np.uint32))
    chunk = 1 << 27
    for start in range(0, top + 1, chunk):
        n = min(chunk, top + 1 - start)
        say("encode patterns", hex(start), n)
        f = np.arange(start, start + n, dtype=np.uint32).view(np.float32)
        got = _gpu_encode(f)
        ref = oracle.e4m3_encode(f)
        if not np.array_equal(got, ref):
            i = np.nonzero(got != ref)[0][:5]
            raise AssertionError([(hex(int(f.view(np.uint32)[j])), float(f[j]), got[j], ref[j]) for j in i])


def test_encode_negative_ragged_and_saturating():
    top = int(np.float32(448.0).view(np.uint32))
    bits = np.arange(0, top + 1, 5, dtype=np.uint32) | np.uint32(0x80000000)
    f = bits.view(np.float32)
    say("encode negatives", f.size)
    assert np.array_equal(_gpu_encode(f), oracle.e4m3_encode(f))
    # beyond +-448 the encoder saturates (clamp first); odd length -> ragged tail
    big = np.array([448.0001, 464, 480, 1e6, 3e38, -448.0001, -500, -3e38, 447.9, -0.0, 0.0],
                   dtype=np.float32)
    got = _gpu_encode(big)
    ref = oracle.e4m3_encode(np.clip(big, -448, 448))
    assert np.array_equal(got, ref)
    assert list(got[:8]) == [0x7E] * 5 + [0xFE] * 3


def _gpu_group_quant(xbits: np.ndarray, ue8m0: bool):
    xd = to_dev_bf16(xbits)
    q, s = fb.quantize_activations(xd, ue8m0=ue8m0)
    return host(q), host(s)


def _golden_groups():
    path = os.path.join(os.path.dirname(__file__), "golden", "group_quant_hand_worked.txt")
    cases, cur = [], None
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *rest = line.split()
        if key == "case":
            cur = {"name": rest[0], "ue8m0": rest[1] == "1"}
            cases.append(cur)
        elif key in ("x", "q"):
            cur[key] = rest
        else:
            cur[key] = rest[0]
    return cases


@pytest.mark.parametrize("case", _golden_groups(), ids=lambda c: c["name"])
def test_group_quant_golden(case):
    x = np.full(128, float(case["fill"]), dtype=np.float32)
    x[: len(case["x"])] = [float(v) for v in case["x"]]
    bits = synth.to_bf16_bits(x)[None, :]
    say("golden", case["name"])
    q, s = _gpu_group_quant(bits, case["ue8m0"])
    if "s_bits" in case:
        assert s[0, 0].view(np.uint32) == int(case["s_bits"], 16)
    else:
        assert s[0, 0] == np.float32(float(case["s"]))
    exp_q = [int(c, 16) for c in case["q"]]
    assert list(q[0, : len(exp_q)]) == exp_q
    assert np.all(q[0, len(exp_q):] == int(case["qfill"], 16))


def test_group_quant_every_bf16_value():
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = (allbits.astype(np.uint32) << 16).view(np.float32)
    finite = np.isfinite(vals)
    rows = []
    for amax in (448.0, 1.0, 3.0e-3, 2.0 ** 100, 1.5 * 2.0 ** -120, 0.0, 3.0e38):
        amax = np.float32(amax)
        keep = allbits[finite & (np.abs(vals) <= amax)] if amax > 0 else allbits[finite & (vals == 0)]
        ng = -(-keep.size // 127)
        groups = np.empty((ng, 128), dtype=np.uint16)
        groups[:, 0] = synth.to_bf16_bits(np.array([amax], np.float32))[0]
        groups[:, 1:] = np.resize(keep, ng * 127).reshape(ng, 127)
        rows.append(groups)
    g = np.concatenate(rows)
    g = np.concatenate([g, np.zeros(((-len(g)) % 8, 128), dtype=np.uint16)])
    x = g.reshape(-1, 8 * 128)  # 8 groups per row
    for ue in (False, True):
        say("every bf16 value, ue8m0", ue, x.shape)
        q, s = _gpu_group_quant(x, ue)
        rq, rs = oracle.group_quant(x, ue8m0=ue)
        assert np.array_equal(s, rs) and np.array_equal(q, rq)


def _quant_cases():
    """The activation operand of every workload once per (M, K): C1-C4, and the
    105 standalone quantizer cases of the C5 sweep (15 M x 7 K)."""
    seen, out = set(), []
    for config in ("single", "decode_8b", "prefill_8b", "ue8m0_32b", "sweep"):
        for c in synth.cases(config):
            key = (config, c.M, c.K)
            if key not in seen:
                seen.add(key)
                out.append(c)
    assert sum(1 for k in seen if k[0] == "sweep") == 105
    return out


@pytest.mark.parametrize("case", _quant_cases(), ids=lambda c: f"{c.config}-M{c.M}-K{c.K}")
def test_group_quant_workloads(case):
    x = synth.activations_bf16(case)
    say("group quant", case.cid, "ue8m0", case.ue8m0)
    q, s = _gpu_group_quant(x, case.ue8m0)
    rq, rs = oracle.group_quant(x, ue8m0=case.ue8m0)
    assert np.array_equal(s, rs), "scales differ"
    if not np.array_equal(q, rq):
        bad = np.argwhere(q != rq)[:5]
        raise AssertionError([(tuple(i), q[tuple(i)], rq[tuple(i)]) for i in bad])


def test_group_quant_strided_and_padding_untouched():
    import torch
    case = synth.Case("decode_8b", "x", 37, 128, 1152, "normal_outlier", False, 0)
    x = synth.activations_bf16(case)
    big = np.zeros((37, 1152 + 64), dtype=np.uint16)
    big[:, :1152] = x
    xd = to_dev_bf16(big)[:, :1152]
    q = torch.full((37, 1152 + 48), 0xAB, dtype=torch.uint8, device=dev())
    s = torch.full((37, 9 + 3), -1.0, dtype=torch.float32, device=dev())
    for ue in (False, True):
        say("strided quant ue8m0", ue)
        fb.fp8_group_quant(xd, q[:, :1152], s[:, :9], ue8m0=ue)
        rq, rs = oracle.group_quant(x, ue8m0=ue)
        qh, sh = host(q), host(s)
        assert np.array_equal(qh[:, :1152], rq) and np.array_equal(sh[:, :9], rs)
        assert np.all(qh[:, 1152:] == 0xAB) and np.all(sh[:, 9:] == -1.0)


def test_group_quant_edges():
    import torch
    # M = 0 is a no-op
    x = torch.empty((0, 256), dtype=torch.bfloat16, device=dev())
    q, s = fb.quantize_activations(x)
    assert q.shape == (0, 256)
    # one group, all zero, with signed zeros
    bits = np.zeros((1, 128), dtype=np.uint16)
    bits[0, 1::2] = 0x8000
    say("single all-zero group")
    q, s = _gpu_group_quant(bits, False)
    assert np.all(q[0, ::2] == 0) and np.all(q[0, 1::2] == 0x80)
    assert s[0, 0] == np.float32(1e-10) / np.float32(448)


WQ_SHAPES = [(256, 384, False), (256, 384, True), (2048, 2048, False), (4096, 12288, False),
             (51200, 5120, True), (2048, 6144, False)]


@pytest.mark.parametrize("N,K,ue8m0", WQ_SHAPES)
def test_weight_block_quant(N, K, ue8m0):
    w = synth.weights_f32(N, K)
    if N == 256:
        w[3, 5] = 7.5  # an outlier in the first block
        w[200, 300] = -0.0
    say("weight quant", N, K, ue8m0)
    q, s = fb.quantize_weight(to_dev(w), ue8m0=ue8m0)
    q, s = host(q), host(s)
    rq, rs = oracle.weight_block_quant(w, ue8m0=ue8m0) if N == 256 else oracle_weight(N, K, ue8m0)
    assert np.array_equal(s, rs) and np.array_equal(q, rq)


@pytest.mark.parametrize("M,K", [(1, 4096), (37, 1152), (8192, 4096)])
def test_scale_output_formats(M, K):
    """Packed E8M0 scale bytes and MN-major scale layout: the same codes, and
    scales that are the oracle's fp32 scales re-laid out (E8M0 byte = the
    biased exponent of the power-of-two scale)."""
    import torch
    case = synth.Case("sweep", "fmt", M, 128, K, "student_t3", True, 77)
    x = synth.activations_bf16(case)
    q_ref, s_ref = oracle.group_quant(x, ue8m0=True)
    e8_ref = (s_ref.view(np.uint32) >> 23).astype(np.uint8)
    xd = to_dev_bf16(x)
    G = K // 128
    for e8m0 in (False, True):
        for mn in (False, True):
            say("scale format", M, K, "e8m0" if e8m0 else "fp32", "mn" if mn else "row")
            q = torch.empty((M, K), dtype=torch.uint8, device=dev())
            dt = torch.uint8 if e8m0 else torch.float32
            pad = 8
            s = torch.full((G, M + pad) if mn else (M, G + pad), 0x5A if e8m0 else -1.0, dtype=dt, device=dev())
            sv = s[:, :M] if mn else s[:, :G]
            fb.fp8_group_quant(xd, q, sv, ue8m0=True, scale_e8m0=e8m0, scale_mn_major=mn)
            sh = host(s)
            assert np.array_equal(host(q), q_ref)
            want = e8_ref if e8m0 else s_ref
            got = sh[:, :M].T if mn else sh[:, :G]
            assert np.array_equal(got, want)
            padv = sh[:, M:] if mn else sh[:, G:]
            assert np.all(padv == (0x5A if e8m0 else -1.0)), "padding written"


def test_largest_quotients_encode_to_448():
    # Groups whose amax a has RN(a / 448) below a / 448, so that a / s lands
    # just above 448: the quantizers convert without a clamp and must still
    # give 0x7E / 0xFE there (the conversion maps everything below 464 to
    # 448).  Group and per-token quantizers against the oracle.
    sig = (np.arange(128, dtype=np.uint32) | np.uint32(0x3F80)) << 16        # bf16 values in [1, 2)
    cand = np.concatenate([sig.view(np.float32) * np.float32(2.0 ** e) for e in (-7, 0, 6)])
    s = (cand / np.float32(448)).astype(np.float32)
    above = cand[s.astype(np.float64) * 448.0 < cand.astype(np.float64)]
    assert above.size > 20
    G = above.size
    rows = np.zeros((G, 128), np.float32)
    rows[:, 0], rows[:, 1] = above, -above
    rows[:, 2:] = above[:, None] * np.linspace(-0.99, 0.99, 126, dtype=np.float32)[None, :]
    bits = synth.to_bf16_bits(rows)
    assert np.array_equal(synth.to_bf16_bits(above[:, None])[:, 0], bits[:, 0])   # amax exact in bf16
    for ue8m0 in (False, True):
        say("largest quotients", G, ue8m0)
        q, sc = _gpu_group_quant(bits, ue8m0)
        rq, rs = oracle.group_quant(bits, EPS, ue8m0)
        assert np.array_equal(q, rq) and np.array_equal(sc, rs)
        if not ue8m0:
            assert np.all(q[:, 0] == 0x7E) and np.all(q[:, 1] == 0xFE)
        import torch
        qt = torch.empty((G, 128), dtype=torch.uint8, device=dev())
        st = torch.empty((G,), dtype=torch.float32, device=dev())
        fb.fp8_token_quant(to_dev_bf16(bits), qt, st, ue8m0=ue8m0)
        tq, ts = oracle.token_quant(bits, ue8m0=ue8m0)
        assert np.array_equal(host(qt), tq) and np.array_equal(host(st), ts)
