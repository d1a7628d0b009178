"""Seeded synthetic inputs for the FP8 blockwise linear layer.

This module only draws random numbers and defines workload shapes; it holds
none of the quantization or GEMM arithmetic.  The same functions feed the
GPU path (tests, benchmark) and the CPU oracle (tests, CPU baseline), so
both see identical bytes.

Workloads (Qwen3-shaped linear layers; the pages benchmark Qwen3 1.7B-32B
models -- autotuning page, "Performance Evaluation"; RFC page, "Standalone
Kernel Performance"):
  single        M=16, N=K=2048, X ~ N(0,1)
  decode_8b     M in {1,8,32,64} x Qwen3-8B (N,K), X ~ N(0,1) with 1% outlier
                channels scaled x20
  prefill_8b    M=8192 (16 sequences x 512) x Qwen3-8B (N,K), outliers as above
  ue8m0_32b     M in {64,4096} x Qwen3-32B (N,K), outliers, power-of-two scales
  sweep         M in {1,2,...,16384} x Qwen3-1.7B/8B/32B (N,K), X ~ Student-t(3)
Weights are W ~ N(0, 0.02) in fp32 (standard deviation 0.02); the quantized
weights are produced from them by a block quantizer (not here).  The fused
producers take the same activation recipes: RMSNorm input X [M, H] with an
fp32 weight 1 + 0.25 N(0,1); SiLU-and-mul input [M, 2I] = [gate | up] drawn
as one activation matrix of width 2I.

Real checkpoints and the pages' serving datasets are not available; these
synthetic tensors of the same shapes stand in for them.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass

import numpy as np

SEED_BASE = 20261203

# (name, N, K) per Qwen3 model; qkv N = (q heads + 2 kv heads) * 128.
SHAPES_1P7B = (("qkv", 4096, 2048), ("o_proj", 2048, 2048),
               ("gate_up", 12288, 2048), ("down", 2048, 6144))
SHAPES_8B = (("qkv", 6144, 4096), ("o_proj", 4096, 4096),
             ("gate_up", 24576, 4096), ("down", 4096, 12288))
SHAPES_32B = (("qkv", 10240, 5120), ("o_proj", 5120, 8192),
              ("gate_up", 51200, 5120), ("down", 5120, 25600))

CONFIG_INDEX = {"single": 0, "decode_8b": 1, "prefill_8b": 2, "ue8m0_32b": 3, "sweep": 4}


@dataclass(frozen=True)
class Case:
    config: str
    shape_name: str
    M: int
    N: int
    K: int
    x_dist: str          # "normal", "normal_outlier", "student_t3"
    ue8m0: bool
    shape_idx: int       # index of (N, K) inside its config (weight seed)

    @property
    def cid(self) -> str:
        return f"{self.config}-{self.shape_name}-M{self.M}-N{self.N}-K{self.K}"

    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


def cases(config: str) -> list[Case]:
    out = []
    if config == "single":
        out.append(Case("single", "linear", 16, 2048, 2048, "normal", False, 0))
    elif config == "decode_8b":
        for si, (nm, N, K) in enumerate(SHAPES_8B):
            for M in (1, 8, 32, 64):
                out.append(Case(config, nm, M, N, K, "normal_outlier", False, si))
    elif config == "prefill_8b":
        for si, (nm, N, K) in enumerate(SHAPES_8B):
            out.append(Case(config, nm, 8192, N, K, "normal_outlier", False, si))
    elif config == "ue8m0_32b":
        for si, (nm, N, K) in enumerate(SHAPES_32B):
            for M in (64, 4096):
                out.append(Case(config, nm, M, N, K, "normal_outlier", True, si))
    elif config == "sweep":
        allshapes = [("1.7b-" + a, b, c) for a, b, c in SHAPES_1P7B] + \
                    [("8b-" + a, b, c) for a, b, c in SHAPES_8B] + \
                    [("32b-" + a, b, c) for a, b, c in SHAPES_32B]
        for si, (nm, N, K) in enumerate(allshapes):
            for e in range(15):
                out.append(Case(config, nm, 1 << e, N, K, "student_t3", False, si))
    else:
        raise KeyError(config)
    return out


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_BASE, *key])))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (round to nearest even) bit patterns, via torch on the CPU."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def outlier_channels(K: int, config_idx: int, shape_idx: int) -> np.ndarray:
    """round(1% of K) distinct channels, fixed per (config, shape)."""
    n = int(round(0.01 * K))
    return np.sort(_rng(config_idx, shape_idx, 2).choice(K, size=n, replace=False))


ROWS_PER_CHUNK = 256


def _chunked(rows: int, cols: int, key: tuple, fill) -> np.ndarray:
    """[rows, cols] fp32 drawn in fixed 256-row chunks, each from its own
    generator keyed by (key, chunk index): the result does not depend on how
    many threads draw it."""
    out = np.empty((rows, cols), dtype=np.float32)
    chunks = [(r0, min(rows, r0 + ROWS_PER_CHUNK)) for r0 in range(0, rows, ROWS_PER_CHUNK)]

    def work(ci_r):
        ci, (r0, r1) = ci_r
        fill(_rng(*key, ci), out[r0:r1])

    workers = max(1, min(16, os.cpu_count() or 1))
    if len(chunks) == 1 or workers == 1:
        for item in enumerate(chunks):
            work(item)
    else:
        with _cf.ThreadPoolExecutor(workers) as ex:
            list(ex.map(work, enumerate(chunks)))
    return out


def _fill_normal(rng, dst):
    rng.standard_normal(size=dst.shape, dtype=np.float32, out=dst)


def _fill_student_t3(rng, dst):
    dst[...] = rng.standard_t(3.0, size=dst.shape)


def activations_f32(case: Case) -> np.ndarray:
    """X [M, K] in fp32 before the bf16 rounding; one draw per (config, shape, M)."""
    M = case.M
    ci = CONFIG_INDEX[case.config]
    key = (ci, case.shape_idx, 0, M)
    if case.x_dist == "student_t3":
        x = _chunked(M, case.K, key, _fill_student_t3)
    else:
        x = _chunked(M, case.K, key, _fill_normal)
        if case.x_dist == "normal_outlier":
            x[:, outlier_channels(case.K, ci, case.shape_idx)] *= np.float32(20.0)
    return x


def activations_bf16(case: Case) -> np.ndarray:
    """X [M, K] as bf16 bit patterns (uint16)."""
    return to_bf16_bits(activations_f32(case))


def weights_f32(case_or_n, K: int | None = None) -> np.ndarray:
    """W [N, K] ~ N(0, 0.02) in fp32; one draw per (N, K): every workload that
    uses a layer shape sees the same weight, whatever its M."""
    if K is None:
        N, K = case_or_n.N, case_or_n.K
    else:
        N = case_or_n
    w = _chunked(N, K, (7, N, K, 1), _fill_normal)
    w *= np.float32(0.02)
    return w


def norm_weight_f32(H: int) -> np.ndarray:
    """RMSNorm weight [H] in fp32: 1 + 0.25 N(0, 1), one draw per H."""
    w = _rng(8, H).standard_normal(H, dtype=np.float32)
    return (np.float32(1.0) + np.float32(0.25) * w).astype(np.float32)


def uniform_f32(shape, lo: float, hi: float, *key: int) -> np.ndarray:
    return _rng(99, *key).uniform(lo, hi, size=shape).astype(np.float32)


def generator(*key: int) -> np.random.Generator:
    """A seeded generator for test-specific draws (codes, scales, rows)."""
    return _rng(98, *key)
