"""Benchmark of the FP8 blockwise-quantized linear layer on one MI355X.

A step is one pass of the whole hot path over every case of the workload:
for each (M, N, K) case one fp8_linear call -- per-token 1x128 activation
quantization of X (bf16 -> e4m3fn + fp32 scales) and the blockwise-scaled
FP8 GEMM in the dispatched variant (Standard / Split-K / Swap-AB; for Swap-AB
the quantizer runs inside the GEMM), bf16 out.  Weights are quantized once on
the GPU before timing.  Inputs are seeded synthetic tensors resident in HBM
before the timed region starts.

Default workload "qwen3_8b": the Qwen3-8B-shaped layers (qkv, o_proj,
gate_up, down) at M in {1, 8, 32, 64} (decode) and M = 8192 (prefill), the
M = 1..8192 range the metric is quoted on.  The step is captured once into a
HIP graph and replayed (the pages run these kernels under graph replay), and
the weights rotate over three copies so that no case re-reads a weight from
the 256 MB Infinity Cache.

Prints one JSON line.  value = GEMM TFLOP/s of the whole step (all GEMM
flops / step time, quantization time included).  Also reported: per-case
times, quant GB/s, the dominant kernel's roofline, and the CPU oracle timed
on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0   # MI355X dense fp8 matrix peak
PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E
WEIGHT_COPIES = 3


def workload_cases(name: str):
    from fp8_blockwise_quantized_token_amd import synth
    if name == "qwen3_8b":
        dec = synth.cases("decode_8b")
        pre = synth.cases("prefill_8b")
        out = []
        for M in (1, 8, 32, 64):
            out += [c for c in dec if c.M == M]
        return out + pre
    if name in ("single", "decode_8b", "prefill_8b", "ue8m0_32b", "sweep"):
        return synth.cases(name)
    raise SystemExit(f"unknown workload {name}")


def gemm_bytes(c, dynamic: bool = False) -> int:
    M, N, K = c.M, c.N, c.K
    if dynamic:  # per-token / per-channel scales
        return M * K + 4 * M + N * K + 4 * N + 2 * M * N
    return M * K + 4 * M * K // 128 + N * K + 4 * (N // 128) * (K // 128) + 2 * M * N


def quant_bytes(c, dynamic: bool = False) -> int:
    return 2 * c.M * c.K + c.M * c.K + (4 * c.M if dynamic else 4 * c.M * c.K // 128)


def kernel_symbol(cfg, fused: bool = False, M: int = 0, channel: bool = False, N: int = 0) -> str:
    """Name of the GEMM kernel a configuration launches, as rocprofv3 prints it."""
    b = lambda v: "true" if v else "false"
    if cfg.variant == 0:
        wm = {64: 32, 128: 64, 256: 128 if cfg.tile_n == 256 else 64}[cfg.tile_m]
        wn = 32 if cfg.kwaves == 2 else 64
        sm = 2 if channel else cfg.scale_mode & 1  # bit 1 is the activation-scale layout
        split = cfg.split_k > 1
        if split and cfg.split_tail and N:
            # whole rounds only: the launcher runs the unsplit kernel (rounds of
            # 256 CUs x workgroups per CU, one per CU for the largest tiles)
            per_cu = 1 if cfg.tile_m * cfg.tile_n >= 256 * 128 else 2
            split = (-(-M // cfg.tile_m) * (N // cfg.tile_n)) % (256 * per_cu) != 0
        return f"k_gemm_lds<{cfg.tile_m}, {cfg.tile_n}, {wm}, {wn}, {b(split)}, {cfg.stages or 2}, {sm}>"
    fq = 0
    if fused:  # the fused quantizer variant the launcher picks for this M
        fq = 16 if cfg.tile_m > 16 or M > 8 else (1 if M <= 1 else 2 if M <= 2 else 4 if M <= 4 else 8)
    return f"k_gemm_swapab<{cfg.tile_m // 16}, {cfg.tile_n // 16}, {b(cfg.split_k > 1)}, {fq}, {b(channel)}>"


def kernel_sources(symbol: str):
    """The source files a kernel is built from (their hash keys the traffic summary)."""
    if symbol.startswith("k_gemm_lds"):
        return ("gemm_standard.hip", "device_common.hpp")
    if symbol.startswith(("k_group_quant", "k_row_quant")):
        return ("quant.hip", "device_common.hpp")
    if symbol.startswith(("k_rms_norm_quant", "k_silu_mul_quant")):
        return ("fused.hip", "device_common.hpp", "sigmoid_table.inc")
    return ("gemm.hip", "device_common.hpp")


PRODUCER_SYMBOLS = {"rms_norm_per_block_quant": "k_rms_norm_quant<8, 1, true>",  # H = 4096
                    "silu_and_mul_per_block_quant": "k_silu_mul_quant<true, 512>"}  # table path, M = 8192


def source_hash(*names: str) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "fp8_blockwise_quantized_token_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(symbol: str):
    """HBM bytes per launch of a kernel from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, copy-calibrated), if it was taken on the
    current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
    except (OSError, ValueError):
        return None
    ent = data.get("kernels", {}).get(symbol)
    if ent is None or ent.get("source_hash") != source_hash(*kernel_sources(symbol)):
        return None
    return ent.get("bytes_per_launch")


ROTATE_BYTES = 1 << 30  # bytes each timing cycle touches: four times the Infinity Cache
TRIALS = 5
# launches per captured graph in the per-case timing: the same for every case
# (and at least the most rotation copies any case gets), so each case
# dispatches its kernels equally often and a profiler's per-kernel average
# over the run is the mean over cases that the roofline figure uses
GRAPH_LAUNCHES = 64


def rotation_copies(copies, nbytes: int, dev, limit: int = 64):
    """At least ROTATE_BYTES / nbytes (at most limit, at least len(copies))
    device copies of an operand, made by cloning the given ones in turn."""
    want = min(limit, max(len(copies), -(-ROTATE_BYTES // max(nbytes, 1))))
    out = list(copies)
    i = 0
    while len(out) < want:
        out.append(tuple(t.clone() for t in copies[i % len(copies)]))
        i += 1
    return out


def graph_time(stream, launches) -> float:
    """Median over TRIALS replays of one captured graph of the given launches,
    seconds per launch (HIP events on the launch stream)."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for fn in launches:
            fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    with torch.cuda.stream(stream):
        g.replay()
        for _ in range(TRIALS):
            e0.record(stream)
            g.replay()
            e1.record(stream)
            e1.synchronize()
            times.append(e0.elapsed_time(e1) * 1e-3 / len(launches))
    del g
    times.sort()
    return times[len(times) // 2]


def extra_measurements(stream, dev):
    """Two figures beside the step, each timed like the per-case ones:
    the UE8M0 Qwen3-32B layers at M = 4096 (power-of-two scales applied by
    the matrix core) and the standalone quantizer at M = 16384 x K in
    {12288, 25600} from the wide sweep."""
    import numpy as np
    import torch
    import fp8_blockwise_quantized_token_amd as fb
    from fp8_blockwise_quantized_token_amd import synth

    out = {"ue8m0_32b_m4096": [], "quant_m16384": []}
    flags = fb.FLAG_UE8M0 | fb.FLAG_WEIGHT_POW2
    for c in synth.cases("ue8m0_32b"):
        if c.M != 4096:
            continue
        w = torch.from_numpy(synth.weights_f32(c.N, c.K)).to(dev)
        qw, sw = fb.quantize_weight(w, ue8m0=True, stream=stream)
        del w
        x = torch.from_numpy(synth.activations_bf16(c).view(np.int16)).to(dev).view(torch.bfloat16)
        y = torch.empty((c.M, c.N), dtype=torch.bfloat16, device=dev)
        cfg = fb.fp8_block_gemm_select(c.M, c.N, c.K, flags)
        ws = fb.linear_workspace(c.M, c.N, c.K, cfg, dev)
        stream.synchronize()
        wc = rotation_copies([(qw, sw)], c.N * c.K, dev)
        t = graph_time(stream, [lambda r=r: fb.fp8_linear(x, wc[r % len(wc)][0], wc[r % len(wc)][1], y,
                                                          ue8m0=True, cfg=cfg, workspace=ws, stream=stream,
                                                          weight_pow2=True)
                                for r in range(max(len(wc), 8))])
        tf = c.flops() / t / 1e12
        out["ue8m0_32b_m4096"].append({"case": c.cid, "cfg": cfg.as_dict(), "linear_us": round(t * 1e6, 2),
                                       "tflops": round(tf, 1), "mfma_frac": round(tf / PEAK_FP8_TFLOPS, 4)})
        print(f"[bench] {c.cid}: {t * 1e6:.1f} us, {tf:.0f} TFLOP/s", file=sys.stderr, flush=True)
        del x, y, ws, wc, qw, sw
    for c in synth.cases("sweep"):
        if c.M != 16384 or c.K not in (12288, 25600) or c.N not in (4096, 5120):
            continue
        x = torch.from_numpy(synth.activations_bf16(c).view(np.int16)).to(dev).view(torch.bfloat16)
        q = torch.empty((c.M, c.K), dtype=torch.uint8, device=dev)
        s = torch.empty((c.M, c.K // 128), dtype=torch.float32, device=dev)
        xc = rotation_copies([(x,)], 2 * c.M * c.K, dev)
        oc = [(q, s)] + [(torch.empty_like(q), torch.empty_like(s)) for _ in range(len(xc) - 1)]
        t = graph_time(stream, [lambda r=r: fb.fp8_group_quant(xc[r % len(xc)][0], oc[r % len(oc)][0],
                                                                oc[r % len(oc)][1], stream=stream)
                                for r in range(max(len(xc), 4))])
        gbps = quant_bytes(c) / t / 1e9
        out["quant_m16384"].append({"M": c.M, "K": c.K, "us": round(t * 1e6, 2), "gbps": round(gbps, 1),
                                    "hbm_frac": round(gbps / PEAK_HBM_GBPS, 4)})
        print(f"[bench] quant {c.M}x{c.K}: {t * 1e6:.1f} us, {gbps:.0f} GB/s", file=sys.stderr, flush=True)
        del x, q, s, xc, oc
    torch.cuda.empty_cache()
    return out


def trace_from_profiles(symbol: str):
    """The rocprofv3 average duration (us) of a kernel from the committed
    kernel-trace summary, if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", "kernel_trace.json")
    try:
        ent = json.load(open(path)).get("kernels", {}).get(symbol)
    except (OSError, ValueError):
        return None
    if ent is None or ent.get("source_hash") != source_hash(*kernel_sources(symbol)):
        return None
    return ent.get("avg_us")


def cpu_baseline(cases, xs, budget_s: float, dynamic: bool = False):
    """The oracle (untuned) on a bounded sample: every case's quantization and
    fp64 GEMM on its first rows, doubling the rows until one pass takes
    about half the budget (or every row of every case is covered)."""
    import numpy as np
    import oracle
    from fp8_blockwise_quantized_token_amd import synth

    threads = oracle.default_threads()
    wcache = {}
    for c in cases:
        key = (c.N, c.K, c.ue8m0)
        if key not in wcache:
            w = synth.weights_f32(c.N, c.K)
            wcache[key] = (oracle.channel_quant(w, ue8m0=c.ue8m0) if dynamic else
                           oracle.weight_block_quant(w, ue8m0=c.ue8m0, nthreads=threads))
    nrows = 1
    while True:
        f = 0.0
        r_used = 0
        t_total = 0.0
        for c, x in zip(cases, xs):
            r = min(nrows, c.M)
            qw, sw = wcache[(c.N, c.K, c.ue8m0)]
            rows = np.ascontiguousarray(x[:r])
            t0 = time.perf_counter()
            if dynamic:
                qa, sa = oracle.token_quant(rows, ue8m0=c.ue8m0, nthreads=threads)
                oracle.scaled_mm(qa, sa, qw, sw, nthreads=threads)
            else:
                qa, sa = oracle.group_quant(rows, ue8m0=c.ue8m0, nthreads=threads)
                oracle.block_gemm(qa, sa, qw, sw, nthreads=threads)
            t_total += time.perf_counter() - t0
            f += 2.0 * r * c.N * c.K
            r_used += r
        if t_total > budget_s / 2 or all(nrows >= c.M for c in cases):
            break
        nrows *= 2
    return {"value": round(f / t_total / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"first min(M, {nrows}) rows of each of the {len(cases)} cases ({r_used} rows, "
                      f"{f / 1e9:.1f} GFLOP; oracle quantizer + fp64 GEMM), {t_total:.1f} s on "
                      f"{threads} host threads"}


PRODUCER_M = (1, 8, 32, 64, 8192)
PRODUCER_H, PRODUCER_I = 4096, 12288  # Qwen3-8B hidden and intermediate sizes


def producer_bytes(op: str, M: int) -> int:
    """Algorithmic HBM bytes of one call: inputs read once, outputs written once."""
    if op == "rms_norm_per_block_quant":
        H = PRODUCER_H
        return 2 * M * H + 4 * H + M * H + 4 * M * H // 128
    I = PRODUCER_I
    return 4 * M * I + M * I + 4 * M * I // 128


def bench_producers(args) -> int:
    """The fused producers of the GEMM's activation operand at Qwen3-8B sizes:
    each call timed by replaying a graph of kernel_reps launches, HIP events
    on the launch stream.  value = algorithmic GB/s over all cases."""
    import torch
    import numpy as np
    import fp8_blockwise_quantized_token_amd as fb
    import oracle
    from fp8_blockwise_quantized_token_amd import synth

    fb.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream()
    w = torch.from_numpy(synth.norm_weight_f32(PRODUCER_H)).to(dev)
    cases = []
    for op in ("rms_norm_per_block_quant", "silu_and_mul_per_block_quant"):
        for M in PRODUCER_M:
            K = PRODUCER_H if op.startswith("rms") else 2 * PRODUCER_I
            xh = synth.activations_bf16(synth.Case("prefill_8b", "producer", M, 128, K, "normal_outlier",
                                                   False, 7))
            x = torch.from_numpy(xh.view(np.int16)).to(dev).view(torch.bfloat16)
            Ko = K if op.startswith("rms") else K // 2
            q = torch.empty((M, Ko), dtype=torch.uint8, device=dev)
            s = torch.empty((M, Ko // 128), dtype=torch.float32, device=dev)
            if op.startswith("rms"):
                fn = (lambda x=x, q=q, s=s: fb.fp8_rms_norm_per_block_quant(x, w, q, s, stream=stream))
            else:
                fn = (lambda x=x, q=q, s=s: fb.fp8_silu_and_mul_per_block_quant(x, q, s, stream=stream))
            cases.append((op, M, xh, fn))
    torch.cuda.synchronize()
    rows = []
    tot_b = tot_t = 0.0
    for op, M, _, fn in cases:
        with torch.cuda.stream(stream):
            for _ in range(args.warmup):
                fn()
        stream.synchronize()
        # rotate over copies of x so that every cycle reads >= 1 GiB, and
        # over as many output buffers: a buffer rewritten by every launch
        # stays in the Infinity Cache, and its writes never reach HBM
        x0, q0, s0 = fn.__defaults__[:3]
        xs_rot = rotation_copies([(x0,)], x0.numel() * 2, dev)
        out_rot = [(q0, s0)] + [(torch.empty_like(q0), torch.empty_like(s0)) for _ in range(len(xs_rot) - 1)]
        t = graph_time(stream, [lambda r=r: fn(x=xs_rot[r % len(xs_rot)][0], q=out_rot[r % len(out_rot)][0],
                                               s=out_rot[r % len(out_rot)][1])
                                for r in range(max(len(xs_rot), args.kernel_reps))])
        del xs_rot, out_rot
        b = producer_bytes(op, M)
        tot_b += b
        tot_t += t
        rows.append({"op": op, "M": M, "us": round(t * 1e6, 2), "gbps": round(b / t / 1e9, 1),
                     "hbm_frac": round(b / t / 1e9 / PEAK_HBM_GBPS, 4)})
        print(f"[bench] {op} M={M}: {t * 1e6:.2f} us, {b / t / 1e9:.0f} GB/s", file=sys.stderr, flush=True)
    big = [r for r in rows if r["M"] == max(PRODUCER_M)]
    out = {"metric": "fused producer GB/s (rms_norm / silu_and_mul + 1x128 group quant), Qwen3-8B sizes",
           "value": round(tot_b / tot_t / 1e9, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16-in/fp32-compute/e4m3-out", "data": "synthetic (seeded)",
           "config": {"workload": "producers_qwen3_8b", "H": PRODUCER_H, "I": PRODUCER_I,
                      "m_values": list(PRODUCER_M), "graph_replay": True,
                      "timing": "graph replays rotating >= 1 GiB of input copies and as many output buffers, median of 5"},
           "roofline": [{"bound": "hbm", "op": r["op"], "kernel": PRODUCER_SYMBOLS[r["op"]],
                         "achieved": r["gbps"], "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                         "frac": r["hbm_frac"], "avg_launch_us": r["us"],
                         "algorithmic_bytes_per_launch": producer_bytes(r["op"], r["M"]),
                         "traffic": traffic_from_profiles(PRODUCER_SYMBOLS[r["op"]])} for r in big],
           "cases": rows}
    if not args.no_cpu_baseline:
        t_cpu = b_cpu = 0.0
        for op, M, xh, _ in cases:
            r = min(M, 256)
            t0 = time.perf_counter()
            if op.startswith("rms"):
                oracle.rms_norm_per_block_quant(xh[:r], synth.norm_weight_f32(PRODUCER_H))
            else:
                oracle.silu_and_mul_per_block_quant(xh[:r])
            t_cpu += time.perf_counter() - t0
            b_cpu += producer_bytes(op, r)
        out["cpu_baseline"] = {"value": round(b_cpu / t_cpu / 1e9, 3), "unit": "GB/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"first min(M, 256) rows of each case, {t_cpu:.1f} s on 1 host thread"}
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3_8b")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of graph replay")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=24.0)
    ap.add_argument("--kernel-reps", type=int, default=10)
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the UE8M0 32B M=4096 layers and the M=16384 quantizer figures")
    ap.add_argument("--format", choices=("block", "dynamic"), default="block",
                    help="block: Block_FP8 (1x128 / 128x128 scales, the default); "
                         "dynamic: FP8_Dynamic (per-token / per-channel scales)")
    ap.add_argument("--op", choices=("linear", "producers"), default="linear",
                    help="linear: the FP8 linear layer (default); producers: the fused "
                         "rms_norm / silu_and_mul group-quant producers")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): the library has no "
              "multi-GPU path.", file=sys.stderr)
        return 2
    if args.op == "producers":
        return bench_producers(args)

    import torch
    import numpy as np
    import fp8_blockwise_quantized_token_amd as fb
    from fp8_blockwise_quantized_token_amd import synth

    fb.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream()
    cases = workload_cases(args.workload)
    print(f"[bench] workload {args.workload}: {len(cases)} cases", file=sys.stderr, flush=True)

    dynamic = args.format == "dynamic"
    # weights: quantized on the GPU, WEIGHT_COPIES buffers per shape
    wq = {}
    with torch.cuda.stream(stream):
        for c in cases:
            key = (c.N, c.K, c.ue8m0)
            if key in wq:
                continue
            w = torch.from_numpy(synth.weights_f32(c.N, c.K)).to(dev)
            copies = []
            for _ in range(WEIGHT_COPIES):
                q = torch.empty((c.N, c.K), dtype=torch.uint8, device=dev)
                if dynamic:
                    s = torch.empty((c.N,), dtype=torch.float32, device=dev)
                    fb.fp8_weight_channel_quant(w, q, s, ue8m0=c.ue8m0, stream=stream)
                else:
                    s = torch.empty((c.N // 128, c.K // 128), dtype=torch.float32, device=dev)
                    fb.fp8_weight_block_quant(w, q, s, ue8m0=c.ue8m0, stream=stream)
                copies.append((q, s))
            wq[key] = copies
            del w
    stream.synchronize()

    # per-case buffers
    bufs = []
    xs = []
    for i, c in enumerate(cases):
        xh = synth.activations_bf16(c)
        xs.append(xh)
        x = torch.from_numpy(xh.view(np.int16)).to(dev).view(torch.bfloat16)
        qa = torch.empty((c.M, c.K), dtype=torch.uint8, device=dev)
        # block format: token-contiguous activation scales, as fp8_linear lays
        # them out for its GEMM
        sa = torch.empty((c.M,) if dynamic else (c.K // 128, c.M), dtype=torch.float32, device=dev)
        y = torch.empty((c.M, c.N), dtype=torch.bfloat16, device=dev)
        cfg = fb.fp8_block_gemm_select(c.M, c.N, c.K, (fb.FLAG_UE8M0 | fb.FLAG_WEIGHT_POW2) if c.ue8m0 else 0)
        gcfg = cfg if dynamic else fb.make_config(cfg.variant, cfg.tile_m, cfg.tile_n, cfg.split_k, cfg.kwaves,
                                                  cfg.stages, cfg.scale_mode | fb.SCALES_SA_MN_MAJOR,
                                                  cfg.split_tail)
        ws = fb.workspace_for(c.M, c.N, c.K, cfg, dev)
        lws = fb.linear_workspace(c.M, c.N, c.K, cfg, dev)
        qw, sw = wq[(c.N, c.K, c.ue8m0)][i % WEIGHT_COPIES]
        bufs.append(dict(case=c, x=x, qa=qa, sa=sa, y=y, cfg=cfg, gcfg=gcfg, ws=ws, lws=lws, qw=qw, sw=sw,
                         fused=cfg.variant == fb.SWAPAB and not dynamic
                         and (cfg.tile_m <= 32 or (cfg.tile_m == 64 and cfg.tile_n == 16))))
    torch.cuda.synchronize()

    def quant(b, x=None, out=None):
        x = b["x"] if x is None else x
        qa, sa = (b["qa"], b["sa"]) if out is None else out
        if dynamic:
            fb.fp8_token_quant(x, qa, sa, ue8m0=b["case"].ue8m0, stream=stream)
        else:
            fb.fp8_group_quant(x, qa, sa, ue8m0=b["case"].ue8m0, stream=stream, scale_mn_major=True)

    def gemm(b, w=None):
        qw, sw = (b["qw"], b["sw"]) if w is None else w
        if dynamic:
            fb.fp8_scaled_mm(b["qa"], b["sa"], qw, sw, b["y"], b["cfg"], b["ws"], stream=stream)
        else:
            fb.fp8_block_gemm(b["qa"], b["sa"], qw, sw, b["y"], b["gcfg"], b["ws"], stream=stream)

    def linear(b, w=None):
        qw, sw = (b["qw"], b["sw"]) if w is None else w
        if dynamic:  # FP8_Dynamic: per-token quantization, then scaled_mm
            quant(b)
            fb.fp8_scaled_mm(b["qa"], b["sa"], qw, sw, b["y"], b["cfg"], b["ws"], stream=stream)
        else:
            fb.fp8_linear(b["x"], qw, sw, b["y"], ue8m0=b["case"].ue8m0, cfg=b["cfg"],
                          workspace=b["lws"], stream=stream, weight_pow2=b["case"].ue8m0)

    def step():
        for b in bufs:
            linear(b)

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step()
    stream.synchronize()

    graph = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            step()
        graph.replay()
        stream.synchronize()

    # ---- timed region: K steps ----
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    ev0.record(stream)
    with torch.cuda.stream(stream):
        for _ in range(args.steps):
            if graph is not None:
                graph.replay()
            else:
                step()
    ev1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_per_step = ev0.elapsed_time(ev1) / args.steps

    total_flops = sum(b["case"].flops() for b in bufs)
    value = total_flops / (ms_per_step * 1e-3) / 1e12

    # ---- per-case and per-kernel durations ----
    # Every case is timed from a captured graph of launches replayed TRIALS
    # times (median), HIP events on the launch stream.  The launches rotate
    # over enough copies of the weight (and, for the quantizer, of X and of
    # its outputs) that each cycle touches at least ROTATE_BYTES, so no launch
    # finds its operand in the 256 MB Infinity Cache, nor writes into a
    # buffer the previous launch left there (a GEMM's output is not rotated:
    # measured 0.5 % on the prefill layers).  quant: fp8_group_quant alone;
    # gemm: the GEMM kernel of the step's call (fused Swap-AB: fp8_linear
    # itself; otherwise fp8_block_gemm on the quantized input; a split-K call
    # includes its reduce kernel); linear: the step's fp8_linear call.
    per_case = []
    sym_time = {}
    sym_work = {}
    for b in bufs:
        c = b["case"]
        wcopies = rotation_copies(wq[(c.N, c.K, c.ue8m0)], c.N * c.K, dev, limit=GRAPH_LAUNCHES)
        xcopies = rotation_copies([(b["x"],)], 2 * c.M * c.K, dev, limit=8)
        qcopies = [(torch.empty_like(b["qa"]), torch.empty_like(b["sa"])) for _ in xcopies]
        nq = max(len(xcopies), 8)
        tq = graph_time(stream, [lambda r=r: quant(b, x=xcopies[r % len(xcopies)][0],
                                                   out=qcopies[r % len(qcopies)]) for r in range(nq)])
        lin = [lambda r=r: linear(b, w=wcopies[r % len(wcopies)]) for r in range(GRAPH_LAUNCHES)]
        tl = graph_time(stream, lin)
        if b["fused"]:
            tg = tl
        else:
            quant(b)
            tg = graph_time(stream, [lambda r=r: gemm(b, w=wcopies[r % len(wcopies)])
                                     for r in range(GRAPH_LAUNCHES)])
        del wcopies, xcopies, qcopies
        fl = c.flops()
        gb = gemm_bytes(c, dynamic) + (2 * c.M * c.K - c.M * c.K - 4 * c.M * c.K // 128 if b["fused"] else 0)
        lb = gemm_bytes(c, dynamic) + quant_bytes(c, dynamic) if not b["fused"] else gb
        sym = kernel_symbol(b["cfg"], b["fused"], c.M, dynamic, c.N)
        sym_time[sym] = sym_time.get(sym, 0.0) + tg
        w = sym_work.setdefault(sym, [0.0, 0.0, 0, 0])
        w[0] += fl
        w[1] += gb
        w[2] += 1
        w[3] += 1 if b["cfg"].split_k > 1 else 0
        roof_t = max(fl / (PEAK_FP8_TFLOPS * 1e12), gb / (PEAK_HBM_GBPS * 1e9))
        per_case.append({
            "case": c.cid, "cfg": b["cfg"].as_dict(), "kernel": sym,
            "linear_us": round(tl * 1e6, 2), "gemm_us": round(tg * 1e6, 2), "quant_us": round(tq * 1e6, 2),
            "gemm_tflops": round(fl / tg / 1e12, 2), "gemm_gbps": round(gb / tg / 1e9, 1),
            "gemm_roofline_frac": round(roof_t / tg, 4),
            "linear_tflops": round(fl / tl / 1e12, 2), "linear_gbps": round(lb / tl / 1e9, 1),
            "quant_gbps": round(quant_bytes(c, dynamic) / tq / 1e9, 1),
        })
        print(f"[bench] {c.cid}: linear {tl * 1e6:.2f} us, gemm {tg * 1e6:.2f} us, quant {tq * 1e6:.2f} us",
              file=sys.stderr, flush=True)

    dom = max(sym_time, key=sym_time.get)
    dflops, dbytes, dlaunches, dsplit = sym_work[dom]
    avg_t = sym_time[dom] / dlaunches
    flop_per_launch = dflops / dlaunches
    byte_per_launch = dbytes / dlaunches
    mfma_bound = flop_per_launch / (PEAK_FP8_TFLOPS * 1e12) >= byte_per_launch / (PEAK_HBM_GBPS * 1e9)
    traffic = traffic_from_profiles(dom)
    if mfma_bound:
        ach = flop_per_launch / avg_t / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / PEAK_FP8_TFLOPS, 4), "traffic": traffic}
    else:
        ach = byte_per_launch / avg_t / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBPS, 4), "traffic": traffic}
    roof["kernel"] = dom
    roof["avg_launch_us"] = round(avg_t * 1e6, 2)
    # the same kernel's average under rocprofv3 --kernel-trace (committed
    # summary of a profiled bench.py run on the current sources), and the
    # fraction of peak it implies
    rp = trace_from_profiles(dom)
    roof["rocprof_avg_launch_us"] = round(rp, 2) if rp else None
    if rp:
        w_ = flop_per_launch / (rp * 1e-6) / 1e12 if mfma_bound else byte_per_launch / (rp * 1e-6) / 1e9
        roof["frac_rocprof"] = round(w_ / (PEAK_FP8_TFLOPS if mfma_bound else PEAK_HBM_GBPS), 4)
    else:
        roof["frac_rocprof"] = None
    roof["launches_measured"] = dlaunches
    roof["timing"] = ("HIP events over graph replays of back-to-back launches rotating >= 1 GiB of weight "
                      "copies, median of 5")
    roof["algorithmic_per_launch"] = {"flop": flop_per_launch, "bytes": byte_per_launch}
    if dsplit:
        roof["note"] = "split-K calls: duration includes the reduce kernel"

    qb = sum(quant_bytes(b["case"], dynamic) for b in bufs)
    qt = sum(p["quant_us"] for p in per_case) * 1e-6
    dec = [(p, b) for p, b in zip(per_case, bufs) if b["case"].M <= 64]
    dec_bytes = sum(gemm_bytes(b["case"], dynamic) for _, b in dec)
    dec_t = sum(p["linear_us"] for p, _ in dec) * 1e-6
    pre = [(p, b) for p, b in zip(per_case, bufs) if b["case"].M >= 4096]
    pre_fl = sum(b["case"].flops() for _, b in pre)
    pre_t = sum(p["linear_us"] for p, _ in pre) * 1e-6

    out = {
        "metric": "FP8 block GEMM TFLOP/s + quant GB/s at M=1..8192, % of MI355X roofline",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3-in/fp32-acc/bf16-out",
        "data": "synthetic (seeded; Qwen3-shaped layers, random weights N(0,0.02))",
        "config": {"workload": args.workload, "cases": len(cases),
                   "m_values": sorted({b["case"].M for b in bufs}),
                   "nk": sorted({(b["case"].N, b["case"].K) for b in bufs}),
                   "format": args.format,
                   "call": "fp8_token_quant + fp8_scaled_mm" if dynamic else "fp8_linear",
                   "graph_replay": graph is not None,
                   "weight_copies": WEIGHT_COPIES},
        "quant_gbps": round(qb / qt / 1e9, 1) if qt > 0 else None,
        "decode_linear_gbps": round(dec_bytes / dec_t / 1e9, 1) if dec_t > 0 else None,
        "prefill_linear_tflops": round(pre_fl / pre_t / 1e12, 1) if pre_t > 0 else None,
        "roofline": roof,
        "cases": per_case,
        "wall_s_timed": round(t_wall, 3),
    }
    if not args.no_extra and args.workload == "qwen3_8b" and not dynamic:
        del bufs
        torch.cuda.empty_cache()
        out["extra"] = extra_measurements(stream, dev)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(cases, xs, args.cpu_budget, dynamic)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
