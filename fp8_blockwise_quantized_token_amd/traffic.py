"""HBM traffic per kernel launch from rocprofv3 counters (run on an MI355X).

Two steps, each under its own rocprofv3 counter pass:

  rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir_f> -o p -- \\
      python3 fp8_blockwise_quantized_token_amd/traffic.py run
  rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir_w> -o p -- \\
      python3 fp8_blockwise_quantized_token_amd/traffic.py run
  python3 fp8_blockwise_quantized_token_amd/traffic.py summarize <dir_f> <dir_w> \\
      --out profiles/hbm_traffic.json

``run`` launches every case of the workload once through fp8_linear (and
once through fp8_block_gemm on pre-quantized input with token-contiguous
scales, as fp8_linear lays them out, so the Standard GEMM kernel is seen
alone), the two fused producers at the producer benchmark's largest size,
plus a plain device-to-device copy of a known size.

``trace`` records the per-kernel average durations of a rocprofv3
``--kernel-trace --stats`` run of bench.py (its ``*kernel_stats.csv``),
keyed by kernel name and source hash like the traffic, so that bench.py can
print the profiler's figure for its dominant kernel beside its own:

  rocprofv3 --kernel-trace --stats --output-format csv -d <dir_t> -o p -- python3 bench.py ...
  python3 fp8_blockwise_quantized_token_amd/traffic.py trace <dir_t> --out profiles/kernel_trace.json
``summarize`` averages FETCH_SIZE and WRITE_SIZE (KiB per dispatch) per
kernel, scales each by what the same counter reads for the copy (bytes
expected / bytes counted), and records the result keyed by the kernel name
and by a hash of the kernel sources, so a reader can tell when the numbers
no longer describe the code.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

COPY_BYTES = 1 << 30
PREFIX = "fp8blk::(anonymous namespace)::"


def _bench():
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import bench
    return bench


def short_name(name: str) -> str:
    if name.startswith("void "):
        name = name[len("void "):]
    if name.startswith(PREFIX):
        name = name[len(PREFIX):]
    depth = 0
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return name[:i]
    return name


def run(workload: str) -> None:
    import numpy as np
    import torch
    import fp8_blockwise_quantized_token_amd as fb
    from fp8_blockwise_quantized_token_amd import synth
    sys.path.insert(0, ROOT)
    import bench

    dev = torch.device("cuda:0")
    cases = bench.workload_cases(workload)
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    wq = {}
    for c in cases:
        key = (c.N, c.K, c.ue8m0)
        if key not in wq:
            w = torch.from_numpy(synth.weights_f32(c.N, c.K)).to(dev)
            wq[key] = fb.quantize_weight(w, ue8m0=c.ue8m0)
            del w
        qw, sw = wq[key]
        x = torch.from_numpy(synth.activations_bf16(c).view(np.int16)).to(dev).view(torch.bfloat16)
        cfg = fb.fp8_block_gemm_select(c.M, c.N, c.K)
        print(f"[traffic] {c.cid} {cfg.as_dict()}", flush=True)
        fb.linear(x, qw, sw, ue8m0=c.ue8m0, cfg=cfg)
        if cfg.variant == fb.STANDARD:
            qa = torch.empty((c.M, c.K), dtype=torch.uint8, device=dev)
            sa = torch.empty((c.K // 128, c.M), dtype=torch.float32, device=dev)
            fb.fp8_group_quant(x, qa, sa, ue8m0=c.ue8m0, scale_mn_major=True)
            gcfg = fb.make_config(cfg.variant, cfg.tile_m, cfg.tile_n, cfg.split_k, cfg.kwaves, cfg.stages,
                                  cfg.scale_mode | fb.SCALES_SA_MN_MAJOR, cfg.split_tail)
            fb.block_gemm(qa, sa, qw, sw, gcfg)
        torch.cuda.synchronize()
    # the fused producers at the producer benchmark's largest size
    bench = _bench()
    M, H, I = max(bench.PRODUCER_M), bench.PRODUCER_H, bench.PRODUCER_I
    case = synth.Case("prefill_8b", "producer", M, 128, H, "normal_outlier", False, 7)
    x = torch.from_numpy(synth.activations_bf16(case).view(np.int16)).to(dev).view(torch.bfloat16)
    w = torch.from_numpy(synth.norm_weight_f32(H)).to(dev)
    print(f"[traffic] rms_norm_per_block_quant M={M} H={H}", flush=True)
    fb.rms_norm_quant(x, w)
    case = synth.Case("prefill_8b", "producer", M, 128, 2 * I, "normal_outlier", False, 7)
    x = torch.from_numpy(synth.activations_bf16(case).view(np.int16)).to(dev).view(torch.bfloat16)
    print(f"[traffic] silu_and_mul_per_block_quant M={M} I={I}", flush=True)
    fb.silu_and_mul_quant(x)
    torch.cuda.synchronize()


def _read_counter(d: str, counter: str) -> dict:
    """Counter value of every dispatch (summed over the rows rocprofv3 writes
    for it), grouped by kernel short name."""
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    per = {}
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") != counter:
                    continue
                k = (short_name(r["Kernel_Name"]), r.get("Dispatch_Id", ""))
                per[k] = per.get(k, 0.0) + float(r["Counter_Value"])
    out = {}
    for (name, _), v in per.items():
        out.setdefault(name, []).append(v)
    return out


def summarize(dir_f: str, dir_w: str, out_path: str) -> None:
    fetch = _read_counter(dir_f, "FETCH_SIZE")
    write = _read_counter(dir_w, "WRITE_SIZE")
    # the calibration copy is the largest device copy of the run
    copy = [k for k in fetch if "copy" in k.lower()]
    copy_f = max(max(fetch[k]) for k in copy)
    copy_w = max(max(write[k]) for k in copy if k in write)
    expected_kib = COPY_BYTES / 1024
    f_fac = expected_kib / copy_f
    w_fac = expected_kib / copy_w
    bench = _bench()
    kernels = {}
    for name in sorted(set(fetch) & set(write)):
        if not name.startswith("k_"):
            continue
        fb_ = sum(fetch[name]) / len(fetch[name]) * f_fac * 1024
        wb_ = sum(write[name]) / len(write[name]) * w_fac * 1024
        kernels[name] = {"fetch_bytes": round(fb_), "write_bytes": round(wb_),
                         "bytes_per_launch": round(fb_ + wb_), "dispatches": len(fetch[name]),
                         "source_hash": bench.source_hash(*bench.kernel_sources(name))}
    data = {"counters": ["FETCH_SIZE", "WRITE_SIZE"], "unit": "bytes per dispatch (average)",
            "calibration": {"copy_bytes": COPY_BYTES, "copy_kernel": copy,
                            "fetch_kib_read": copy_f, "write_kib_read": copy_w,
                            "fetch_factor": f_fac, "write_factor": w_fac},
            "kernels": kernels}
    with open(out_path, "w") as f:
        json.dump(data, f, indent=1)
    print(json.dumps(data["calibration"]))
    for k, v in kernels.items():
        print(f"{k:60s} fetch {v['fetch_bytes'] / 1e6:10.2f} MB  write {v['write_bytes'] / 1e6:9.2f} MB "
              f"({v['dispatches']} dispatches)")


def trace(dir_t: str, out_path: str, command: str = "") -> None:
    files = glob.glob(os.path.join(dir_t, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {dir_t}")
    bench = _bench()
    kernels = {}
    with open(files[0]) as f:
        for r in csv.DictReader(f):
            name = short_name(r["Name"])
            if not name.startswith("k_"):
                continue
            kernels[name] = {"calls": int(r["Calls"]), "avg_us": float(r["AverageNs"]) / 1e3,
                             "min_us": float(r["MinNs"]) / 1e3, "max_us": float(r["MaxNs"]) / 1e3,
                             "percent": float(r["Percentage"]),
                             "source_hash": bench.source_hash(*bench.kernel_sources(name))}
    with open(out_path, "w") as f:
        json.dump({"unit": "microseconds per dispatch", "command": command, "kernels": kernels}, f, indent=1)
    for k, v in sorted(kernels.items(), key=lambda kv: -kv[1]["percent"])[:12]:
        print(f"{k:60s} {v['calls']:6d} {v['avg_us']:10.2f} us {v['percent']:6.2f} %")


def main() -> int:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("run")
    r.add_argument("--workload", default="qwen3_8b")
    s = sub.add_parser("summarize")
    s.add_argument("dir_fetch")
    s.add_argument("dir_write")
    s.add_argument("--out", default=os.path.join(ROOT, "profiles", "hbm_traffic.json"))
    t = sub.add_parser("trace")
    t.add_argument("dir_trace")
    t.add_argument("--out", default=os.path.join(ROOT, "profiles", "kernel_trace.json"))
    t.add_argument("--command", default="", help="the profiled command, recorded with the figures")
    a = ap.parse_args()
    if a.cmd == "run":
        run(a.workload)
    elif a.cmd == "trace":
        trace(a.dir_trace, a.out, a.command)
    else:
        summarize(a.dir_fetch, a.dir_write, a.out)
    return 0


if __name__ == "__main__":
    sys.exit(main())
