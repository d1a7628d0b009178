"""Offline per-shape tuning of the GEMM configuration (run on an MI355X).

The pages select, per input shape, the best GEMM variant and tile
configuration by ahead-of-time tuning and ship the result as a table
(page "Helion: improving vLLM inference with autotuning", sections "Kernel
Implementation", "Per-shape Config Tuning" and "Enable CUDA Graph for
Autotuner Benchmarking").  This module does the same for libfp8blk: for each
(M, N, K) it times every valid configuration under HIP-graph replay, with the
weights rotated over enough copies that no launch re-reads a weight from the
256 MB Infinity Cache, and records the fastest.  ``--write-table`` turns a
result file into ``csrc/dispatch_table.inc`` (buckets of M keyed on (N, K)).

By default the whole layer is timed (``fp8_linear``: activation quantization
included, fused into the GEMM for Swap-AB configurations), since that is the
call the table serves on the hot path; ``--op gemm`` times
``fp8_block_gemm`` on pre-quantized activations instead.

  python -m fp8_blockwise_quantized_token_amd.tune --shapes all --out tune.json
  python -m fp8_blockwise_quantized_token_amd.tune --write-table tune.json

``--merge-table`` re-tunes part of the table instead: for every result whose
(N, K, M) ends a bucket of the current table, the bucket takes the fastest
configuration when it beats the one dispatched now by more than
``--min-gain`` (timing noise is about 1-2 %); other buckets are kept.

  python -m fp8_blockwise_quantized_token_amd.tune --shapes 8b --ms 32,64 --out part.json
  python -m fp8_blockwise_quantized_token_amd.tune --merge-table part.json
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
if os.path.dirname(HERE) not in sys.path:
    sys.path.insert(0, os.path.dirname(HERE))

M_VALUES = [1, 2, 4, 8, 16, 24, 32, 48, 64, 96, 128, 192, 256, 384, 512, 768, 1024,
            1536, 2048, 3072, 4096, 6144, 8192, 12288, 16384]


def shape_sets(name: str):
    from fp8_blockwise_quantized_token_amd import synth
    sets = {"1.7b": synth.SHAPES_1P7B, "8b": synth.SHAPES_8B, "32b": synth.SHAPES_32B}
    names = list(sets) if name == "all" else name.split(",")
    out = []
    for n in names:
        out += [(N, K) for _, N, K in sets[n]]
    return out


def candidates(M: int, N: int, K: int):
    import fp8_blockwise_quantized_token_amd as fb
    kb = K // 128
    out = []
    if M <= 64:
        tm = 16 if M <= 16 else (32 if M <= 32 else 64)
        for tn in (16, 32, 64):
            if tn == 64 and tm == 64:
                continue
            for kw in (1, 2, 4, 8):
                for sk in (1, 2, 4, 8, 16):
                    if sk * kw <= kb:
                        out.append(fb.make_config(fb.SWAPAB, tm, tn, sk, kw))
    stages = {(64, 64): (2, 3, 4), (64, 128): (2, 3, 4), (128, 128): (2, 3), (256, 128): (2, 3), (128, 256): (2,),
              (256, 256): (2,)}
    for tm, tn in ((64, 64), (64, 128), (128, 128), (256, 128), (128, 256), (256, 256)):
        if N % tn or (tm >= 128 and M <= 32):
            continue
        tiles = -(-M // tm) * (N // tn)
        for sk in (1, 2, 3, 4, 6, 8):
            if sk > 1 and (tiles >= 512 or sk * 2 > kb):
                continue
            for ns in stages[(tm, tn)]:
                if ns > 2 and (tiles * sk >= 2048 or kb // sk < ns):
                    continue  # deep pipelines are for few, short K loops
                out.append(fb.make_config(fb.STANDARD, tm, tn, sk, 1, 0 if ns == 2 else ns))
                # twice the waves for grids of about one workgroup per CU
                if (tm, tn) in ((64, 64), (64, 128), (128, 128)) and tiles * sk <= 1024:
                    out.append(fb.make_config(fb.STANDARD, tm, tn, sk, 2, 0 if ns == 2 else ns))
        # split tail: whole rounds unsplit, the partial last round split
        # (rounds of 256 workgroups for the one-per-CU tiles, else 512)
        rnd = 256 if tm * tn >= 256 * 128 else 512
        if tiles > rnd and tiles % rnd:
            for sk in (2, 3, 4, 6, 8):
                if sk * 2 <= kb and (tiles % rnd) * sk <= 2 * rnd:
                    out.append(fb.make_config(fb.STANDARD, tm, tn, sk, 1, 0, split_tail=1))
    return out


def workspace_bytes(fb, op: str, M: int, N: int, K: int, cfg) -> int:
    if op == "linear":
        return fb.fp8_linear_workspace_size(M, N, K, cfg)
    return fb.fp8_block_gemm_workspace_size(M, N, K, cfg)


def time_config(fb, torch, bufs, cfg, reps: int, op: str) -> float:
    """Microseconds per call: a graph of `reps` calls over rotating weight
    copies, replayed 3 times; the best replay counts."""
    M, N, K = bufs["M"], bufs["N"], bufs["K"]
    n = workspace_bytes(fb, op, M, N, K, cfg)
    ws = bufs["ws_pool"][: max(n, 16)] if n else None
    stream = bufs["stream"]
    copies = bufs["w"]

    def call(i):
        qw, sw = copies[i % len(copies)]
        if op == "linear":
            fb.fp8_linear(bufs["x"], qw, sw, bufs["y"], cfg=cfg, workspace=ws, stream=stream)
        else:
            fb.fp8_block_gemm(bufs["a"], bufs["sa"], qw, sw, bufs["y"], cfg, ws, stream=stream)

    with torch.cuda.stream(stream):
        for i in range(2):
            call(i)
    stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(reps):
            call(i)
    best = float("inf")
    for _ in range(3):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            g.replay()  # replays on the current stream
            e1.record(stream)
        e1.synchronize()
        best = min(best, e0.elapsed_time(e1) * 1e3 / reps)
    del g
    return best


def run_sweep(args) -> dict:
    import numpy as np
    import torch
    import fp8_blockwise_quantized_token_amd as fb

    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream()
    shapes = ([tuple(int(v) for v in nk.split("x")) for nk in args.nk.split(",")] if args.nk
              else shape_sets(args.shapes))
    ms = [int(m) for m in args.ms.split(",")] if args.ms else M_VALUES
    results = {"device": torch.cuda.get_device_name(0), "op": args.op, "entries": []}
    ws_pool = torch.empty((1 << 30,), dtype=torch.uint8, device=dev)  # 1 GiB split-K workspace pool
    t0 = time.time()
    for (N, K) in shapes:
        wbytes = N * K
        ncopies = max(2, min(40, -(-(1 << 30) // wbytes)))
        gen = torch.Generator(device=dev)
        gen.manual_seed(N * 131 + K)
        copies = []
        for _ in range(ncopies):
            qw = torch.randint(0, 256, (N, K), dtype=torch.uint8, device=dev, generator=gen)
            qw[qw == 0x7F] = 0x38
            qw[qw == 0xFF] = 0xB8
            sw = torch.rand((N // 128, K // 128), device=dev, generator=gen) + 0.5
            copies.append((qw, sw))
        for M in ms:
            a = torch.randint(0, 256, (M, K), dtype=torch.uint8, device=dev, generator=gen)
            a[a == 0x7F] = 0x38
            a[a == 0xFF] = 0xB8
            sa = torch.rand((M, K // 128), device=dev, generator=gen) + 0.5
            x = torch.randn((M, K), device=dev, generator=gen).to(torch.bfloat16)
            y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            bufs = dict(M=M, N=N, K=K, a=a, sa=sa, x=x, y=y, w=copies, stream=stream, ws_pool=ws_pool)
            flops = 2.0 * M * N * K
            reps = int(min(50, max(4, 2e-3 / max(flops / 2.0e15, wbytes / 6.0e12))))
            timings = []
            dsel = fb.fp8_block_gemm_select(M, N, K)
            disp = dsel.as_dict()
            cands = candidates(M, N, K)
            if all(c.as_dict() != disp for c in cands):
                cands.append(dsel)  # the current choice is always timed
            for cfg in cands:
                if workspace_bytes(fb, args.op, M, N, K, cfg) > ws_pool.numel():
                    continue
                us = time_config(fb, torch, bufs, cfg, reps, args.op)
                timings.append((us, cfg.as_dict()))
            timings.sort(key=lambda t: t[0])
            disp_us = next((t for t, c in timings if c == disp), None)
            best_us, best = timings[0]
            results["entries"].append({"M": M, "N": N, "K": K, "best": best, "best_us": best_us,
                                       "dispatch": disp, "dispatch_us": disp_us,
                                       "top": [{"us": t, "cfg": c} for t, c in timings[:8]]})
            print(f"[tune] M={M:5d} N={N:5d} K={K:5d} best {best_us:9.2f} us "
                  f"({flops / best_us / 1e6:7.1f} TFLOP/s, "
                  f"{(wbytes + M * K + 2 * M * N) / best_us / 1e3:7.1f} GB/s) {best}  "
                  f"dispatch {disp_us} {disp}  [{time.time() - t0:.0f}s]", flush=True)
            del a, sa, x, y, bufs
        del copies
        torch.cuda.empty_cache()
    return results


def write_table(path: str, out_inc: str) -> None:
    """Bucket the sweep: M in (M_prev, M] of a shape uses the config tuned at M."""
    data = json.load(open(path))
    by_shape: dict = {}
    for e in data["entries"]:
        by_shape.setdefault((e["N"], e["K"]), []).append(e)
    lines = ["// dispatch_table.inc -- per-shape GEMM configurations measured on MI355X",
             "// by fp8_blockwise_quantized_token_amd/tune.py (HIP-graph replay, weights",
             f"// rotated past the Infinity Cache; timed call: {data.get('op', 'gemm')}).",
             "// Entry: {N, K, M_lo, M_hi,",
             "// CFG(variant, tile_m, tile_n, split_k, kwaves), CFGS(..., stages) or",
             "// CFGT(..., stages) (split tail)};",
             "// the first bucket containing M wins.",
             "static const Entry kTable[] = {"]
    for (N, K), ents in sorted(by_shape.items()):
        ents.sort(key=lambda e: e["M"])
        lo = 0
        for e in ents:
            b = e["best"]
            hi = e["M"]
            if e is ents[-1]:
                hi = 2147483647 if b["variant"] == "standard" else e["M"]
            cfg = cfg_text(b)
            lines.append(f"    {{{N}, {K}, {lo + 1}, {hi}, {cfg}}},  // {e['best_us']:.2f} us at M={e['M']}")
            lo = e["M"]
    lines.append("};")
    with open(out_inc, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {out_inc}: {sum(len(v) for v in by_shape.values())} entries")


def cfg_text(b: dict) -> str:
    var = "FP8BLK_SWAPAB" if b["variant"] == "swapab" else "FP8BLK_STANDARD"
    ns = b.get("stages", 0)
    if b.get("split_tail", 0):
        return f"CFGT({var}, {b['tile_m']}, {b['tile_n']}, {b['split_k']}, {b['kwaves']}, {ns})"
    if ns == 0:
        return f"CFG({var}, {b['tile_m']}, {b['tile_n']}, {b['split_k']}, {b['kwaves']})"
    return f"CFGS({var}, {b['tile_m']}, {b['tile_n']}, {b['split_k']}, {b['kwaves']}, {ns})"


def merge_table(path: str, inc: str, min_gain: float) -> None:
    """Replace the buckets of `inc` that end at a re-tuned M with the faster
    configuration; print what changed."""
    import re
    data = json.load(open(path))
    lines = open(inc).read().split("\n")
    pat = re.compile(r"^    \{(\d+), (\d+), (\d+), (\d+), (.*)\},  // .*$")
    where = {}
    for i, ln in enumerate(lines):
        m = pat.match(ln)
        if m:
            where[(int(m.group(1)), int(m.group(2)), int(m.group(4)))] = (i, int(m.group(3)))
    changed = 0
    for e in data["entries"]:
        key = (e["N"], e["K"], e["M"])
        if key not in where or e["dispatch_us"] is None:
            continue
        if e["best"] == e["dispatch"] or e["best_us"] > e["dispatch_us"] * (1.0 - min_gain):
            continue
        i, lo = where[key]
        lines[i] = (f"    {{{e['N']}, {e['K']}, {lo}, {e['M']}, {cfg_text(e['best'])}}},  "
                    f"// {e['best_us']:.2f} us at M={e['M']}")
        changed += 1
        print(f"N={e['N']} K={e['K']} M={e['M']}: {e['dispatch_us']:.2f} -> {e['best_us']:.2f} us  {e['best']}")
    with open(inc, "w") as f:
        f.write("\n".join(lines))
    print(f"{inc}: {changed} buckets changed")


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--shapes", default="all", help="all or a comma list of 1.7b,8b,32b")
    ap.add_argument("--nk", default="", help="weight shapes NxK, comma separated (instead of --shapes)")
    ap.add_argument("--ms", default="", help="comma list of M values (default: the standard set)")
    ap.add_argument("--out", default="tune.json")
    ap.add_argument("--op", choices=("linear", "gemm"), default="linear")
    ap.add_argument("--write-table", metavar="RESULTS", help="write csrc/dispatch_table.inc from a result file")
    ap.add_argument("--merge-table", metavar="RESULTS", help="update the buckets of csrc/dispatch_table.inc "
                    "that end at a re-tuned M")
    ap.add_argument("--min-gain", type=float, default=0.03, help="relative gain a merged bucket must show")
    args = ap.parse_args()
    if args.merge_table:
        merge_table(args.merge_table, os.path.join(HERE, "csrc", "dispatch_table.inc"), args.min_gain)
        return 0
    if args.write_table:
        write_table(args.write_table, os.path.join(HERE, "csrc", "dispatch_table.inc"))
        return 0
    res = run_sweep(args)
    with open(args.out, "w") as f:
        json.dump(res, f, indent=1)
    print(f"wrote {args.out}")
    return 0


if __name__ == "__main__":
    sys.exit(main())
