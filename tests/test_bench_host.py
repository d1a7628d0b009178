"""Host logic of bench.py, checked on the CPU against committed profiler data.

* The kernel name bench.py derives from each qwen3_8b case's dispatched
  configuration (the key it uses to look up profiler figures) is a name the
  profiler actually printed for that workload (profiles/kernel_trace.json,
  a rocprofv3 --kernel-trace of bench.py).
* The profiler figures are returned only while the kernel sources hash to
  the recorded value: a changed source gives None.
* The algorithmic byte counts follow from the tensor shapes.
"""
import json
import os
import shutil
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
import fp8_blockwise_quantized_token_amd as fb  # noqa: E402
from fp8_blockwise_quantized_token_amd import synth  # noqa: E402


def _trace():
    return json.load(open(os.path.join(ROOT, "profiles", "kernel_trace.json")))["kernels"]


def test_case_kernel_names_are_the_profiler_names():
    names = set(_trace())
    for c in bench.workload_cases("qwen3_8b"):
        cfg = fb.fp8_block_gemm_select(c.M, c.N, c.K)
        fused = cfg.variant == fb.SWAPAB and (cfg.tile_m <= 32 or (cfg.tile_m == 64 and cfg.tile_n == 16))
        sym = bench.kernel_symbol(cfg, fused, c.M, False, c.N)
        assert sym in names, (c.cid, sym)


def test_profile_figures_follow_the_source_hash(tmp_path, monkeypatch):
    trace = _trace()
    sym = "k_gemm_lds<256, 256, 128, 64, false, 2, 0>"
    rec = trace[sym]
    cur = bench.source_hash(*bench.kernel_sources(sym))
    if rec["source_hash"] == cur:
        assert bench.trace_from_profiles(sym) == rec["avg_us"]
    # a copy of the tree whose GEMM source differs by one byte
    root = tmp_path / "r"
    shutil.copytree(os.path.join(ROOT, "profiles"), root / "profiles")
    shutil.copytree(os.path.join(ROOT, "fp8_blockwise_quantized_token_amd", "csrc"),
                    root / "fp8_blockwise_quantized_token_amd" / "csrc")
    src = root / "fp8_blockwise_quantized_token_amd" / "csrc" / "gemm_standard.hip"
    src.write_text(src.read_text() + "\n")
    monkeypatch.setattr(bench, "ROOT", str(root))
    assert bench.trace_from_profiles(sym) is None
    assert bench.traffic_from_profiles(sym) is None
    # an unknown kernel has no figures
    monkeypatch.setattr(bench, "ROOT", ROOT)
    assert bench.trace_from_profiles("k_not_a_kernel") is None


def test_algorithmic_bytes():
    c = synth.Case("prefill_8b", "x", 8192, 6144, 4096, "normal", False, 0)
    # A codes + sA + W codes + sW + bf16 Y
    assert bench.gemm_bytes(c) == 8192 * 4096 + 4 * 8192 * 32 + 6144 * 4096 + 4 * 48 * 32 + 2 * 8192 * 6144
    # bf16 X in, codes and one fp32 scale per 128 values out
    assert bench.quant_bytes(c) == 2 * 8192 * 4096 + 8192 * 4096 + 4 * 8192 * 32
    # per-token / per-channel: one scale per row of A and of W
    assert bench.gemm_bytes(c, True) == 8192 * 4096 + 4 * 8192 + 6144 * 4096 + 4 * 6144 + 2 * 8192 * 6144
